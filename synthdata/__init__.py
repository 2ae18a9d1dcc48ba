"""Seeded synthetic inputs for the d20 decoder-only Transformer training step.

This module is shared by the test oracle and by the GPU path's tests and
benchmark.  It only *draws* inputs (token rows, per-token byte lengths,
weights, block activations) and describes the flat parameter layout; it holds
none of the model's arithmetic.

Workload recipe (the pages train on packed 2048-token FineWeb-EDU rows that
compress ~4.8 characters per token -- nanochat speedrun walkthrough,
lyylswood.com, sections "Tokenizer" and "Pretraining"; that corpus is not
available, so these draws stand in for it):

* token ids: finite Zipf law p(id) proportional to (id+1)^-1.1 over the whole
  vocabulary (id = frequency rank), drawn by inverse-CDF sampling in float64;
  each row draws T+1 ids, inputs are the first T and targets the last T
  (next-token prediction over packed rows, no document masking);
* bytes per vocabulary id: 1 + Poisson(3.8), mean 4.8, independent of the id;
* weights: N(0, std) with std = 1/sqrt(fan_in), fan_in = number of input
  features (columns of a row-major [out, in] matrix); the embedding table has
  no fan-in and uses std 1.0;
* block activations and upstream gradients: N(0, 1).

Every draw comes from ``numpy.random.SeedSequence(seed).spawn(4)``:
stream 0 tokens, 1 byte lengths, 2 weights, 3 block activations.
bf16 configurations round every drawn float to bfloat16 (round to nearest,
ties to even) before either side sees it, so both sides start from the same
exact values.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Config", "CONFIGS", "get_config", "param_layout", "param_count",
    "make_tokens", "make_token_bytes", "make_params", "make_block_io",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "round_to_bf16",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    d_ff: int
    vocab: int
    batch: int
    seq_len: int
    dtype: str            # "f32" or "bf16"
    seed: int
    block_only: bool = False
    rope_base: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # depth 2, d 128, 2 x 64 heads, MLP 512, vocab 512, 2 x 64 tokens, fp32
    "tiny": Config("tiny", 2, 128, 2, 64, 512, 512, 2, 64, "f32", 0),
    # depth 4, d 256, 2 x 128 heads, MLP 1024, vocab 4096, 8 x 256 tokens, bf16
    "small": Config("small", 4, 256, 2, 128, 1024, 4096, 8, 256, "bf16", 1),
    # one d20 layer at its real shape, 32 x 2048 tokens, bf16, no embedding/head
    "block": Config("block", 1, 1280, 10, 128, 5120, 0, 32, 2048, "bf16", 2,
                    block_only=True),
    # the full d20 model, 32 x 2048 tokens, bf16
    "d20": Config("d20", 20, 1280, 10, 128, 5120, 65536, 32, 2048, "bf16", 3),
    # d30 (64 x depth channels), 16 x 2048 tokens, bf16
    "d30": Config("d30", 30, 1920, 15, 128, 7680, 65536, 16, 2048, "bf16", 4),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.with_(**overrides) if overrides else cfg


# ---------------------------------------------------------------------------
# flat parameter layout: E [V,d]; per layer Wq, Wk, Wv, Wo [d,d], W1 [F,d],
# W2 [d,F]; U [V,d].  All row-major [out, in].  Block-only: one layer's six.
# ---------------------------------------------------------------------------
LAYER_TENSORS = ("Wq", "Wk", "Wv", "Wo", "W1", "W2")


def param_layout(cfg: Config):
    """Ordered list of (name, layer, rows, cols, offset) in elements."""
    d, F, V = cfg.d_model, cfg.d_ff, cfg.vocab
    shapes = {"Wq": (d, d), "Wk": (d, d), "Wv": (d, d), "Wo": (d, d),
              "W1": (F, d), "W2": (d, F)}
    out, off = [], 0
    if not cfg.block_only:
        out.append(("E", -1, V, d, off)); off += V * d
    for l in range(cfg.n_layer):
        for nm in LAYER_TENSORS:
            r, c = shapes[nm]
            out.append((nm, l, r, c, off)); off += r * c
    if not cfg.block_only:
        out.append(("U", -1, V, d, off)); off += V * d
    return out


def param_count(cfg: Config) -> int:
    name, layer, r, c, off = param_layout(cfg)[-1]
    return off + r * c


# ---------------------------------------------------------------------------
# bf16 storage helpers (data preparation: exact bit-level rounding)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _streams(cfg: Config):
    return np.random.SeedSequence(cfg.seed).spawn(4)


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------
_ZIPF_S = 1.1
_BYTES_LAM = 3.8


def make_tokens(cfg: Config, rows: int | None = None):
    """Token ids (int32 [B,T]) and next-token targets (int32 [B,T]).

    The draw is B x (T+1) ids for the configuration's full batch; ``rows``
    keeps only the first rows, so a smaller run sees the same rows."""
    V, B, T = cfg.vocab, cfg.batch, cfg.seq_len
    rng = np.random.default_rng(_streams(cfg)[0])
    pmf = np.arange(1, V + 1, dtype=np.float64) ** (-_ZIPF_S)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random((B, T + 1))
    ids = np.searchsorted(cdf, u, side="right")
    ids = np.minimum(ids, V - 1).astype(np.int32)
    if rows is not None:
        ids = ids[:rows]
    return np.ascontiguousarray(ids[:, :T]), np.ascontiguousarray(ids[:, 1:])


def make_token_bytes(cfg: Config) -> np.ndarray:
    """Bytes per vocabulary id, int32 [V], 1 + Poisson(3.8)."""
    rng = np.random.default_rng(_streams(cfg)[1])
    return (1 + rng.poisson(_BYTES_LAM, size=cfg.vocab)).astype(np.int32)


def make_params(cfg: Config) -> np.ndarray:
    """Flat float32 parameter vector in the layout of ``param_layout``.

    For bf16 configurations every value is already rounded to bf16, so
    ``f32_to_bf16_bits`` of the result is exact."""
    rng = np.random.default_rng(_streams(cfg)[2])
    out = np.empty(param_count(cfg), dtype=np.float32)
    for name, layer, r, c, off in param_layout(cfg):
        std = 1.0 if name == "E" else 1.0 / np.sqrt(c)
        out[off:off + r * c] = rng.standard_normal(r * c, dtype=np.float32) * np.float32(std)
    if cfg.dtype == "bf16":
        out = round_to_bf16(out)
    return out


def make_block_io(cfg: Config, rows: int | None = None):
    """Block input activations x and upstream gradients dy, float32 [B,T,d]."""
    rng = np.random.default_rng(_streams(cfg)[3])
    B, T, d = cfg.batch, cfg.seq_len, cfg.d_model
    x = rng.standard_normal((B, T, d), dtype=np.float32)
    dy = rng.standard_normal((B, T, d), dtype=np.float32)
    if rows is not None:
        x, dy = x[:rows], dy[:rows]
    if cfg.dtype == "bf16":
        x, dy = round_to_bf16(x), round_to_bf16(dy)
    return np.ascontiguousarray(x), np.ascontiguousarray(dy)


def split_params(cfg: Config, flat: np.ndarray) -> dict:
    """View a flat vector as {"E":..., "U":..., "layers": [{"Wq":...}, ...]}."""
    out = {"layers": [dict() for _ in range(cfg.n_layer)]}
    for name, layer, r, c, off in param_layout(cfg):
        a = flat[off:off + r * c].reshape(r, c)
        if layer < 0:
            out[name] = a
        else:
            out["layers"][layer][name] = a
    return out
