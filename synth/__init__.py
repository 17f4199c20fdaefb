"""Seeded synthetic inputs for the Recurrent Looped Transformer decoder step.

This module fixes shapes, value distributions and random streams, and nothing else: it
holds none of the method's arithmetic. Both the CPU oracle (``oracle/``) and the HIP path
(``stateful_decoding_amd``) consume exactly the arrays produced here.

Workloads follow the shapes the pages describe for the decoder: the ~50M (width 512, six
decoder blocks, window 64) and ~140M (width 768, twelve decoder blocks) scales of the
independent evaluation ("16 per-token recurrence, no quality gain", evaluation narrative),
the 48-layer reference decoder ("RLT Runs 96 Blocks Per Token", reference tied
configuration) and the 1024-4096 token lengths of the extrapolation study. The encoder is
not part of the decoder step, so its outputs ``e_t`` are drawn ``N(0, 1)``: the step's cost
depends only on shapes, and a trained encoder's outputs are unit-RMS as well.

Random streams: every tensor has its own ``numpy`` PCG64 stream keyed by
``SeedSequence([seed, tensor_id])``, so any tensor (or any one sequence's encoder outputs)
can be regenerated alone. bf16 configurations round every matrix and every encoder output
to the nearest bf16 value (ties to even) and keep them as float32 arrays, so both sides
see bit-identical operands.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "RLTConfig", "CONFIGS", "round_bf16", "make_params", "make_encoder_outputs",
    "MATRIX_NAMES", "tensor_id", "VOCAB", "make_head_params", "make_tokens", "make_uniforms",
]

# Vocabulary size of the encoder's embedding and the readout (the pages name none; a power of
# two in the range of common language-model vocabularies).
VOCAB = 32768


@dataclass(frozen=True)
class RLTConfig:
    """Shape and numeric settings of one decoder workload.

    ``window`` is W: the attention window including the current token, so W - 1 past
    entries per layer are retained. ``n_groups`` is G: 1 for memory shared by all decoder
    layers, ``n_layers`` for layer-specific memory.
    """
    name: str
    d: int
    n_heads: int
    head_dim: int
    n_layers: int
    ffn: int
    window: int
    n_groups: int
    alpha: float
    batch: int
    seq_len: int
    dtype: str          # "fp32" or "bf16": storage/operand type of matrices, memory, caches
    sigma: float        # std of every weight matrix
    eps: float = 1e-6   # RMSNorm epsilon

    def replace(self, **kw) -> "RLTConfig":
        return dataclasses.replace(self, **kw)

    @property
    def group_of_layer(self):
        return [0 if self.n_groups == 1 else l for l in range(self.n_layers)]


CONFIGS: dict[str, RLTConfig] = {
    # d=64, 2 heads x 32, 2 blocks, FFN 256, W=4, shared memory, alpha=1, B=2, T=32.
    "tiny_fp32": RLTConfig("tiny_fp32", 64, 2, 32, 2, 256, 4, 1, 1.0, 2, 32, "fp32", 0.02),
    # ~50M scale: d=512, 8 heads x 64, 6 blocks, FFN 2048, W=64, G=1, B=64, T=1024.
    "s50m_bf16": RLTConfig("s50m_bf16", 512, 8, 64, 6, 2048, 64, 1, 1.0, 64, 1024, "bf16", 0.02),
    # ~140M scale: d=768, 12 heads x 64, 12 blocks, FFN 3072, W=128, G=12, B=256, T=1024.
    "s140m_bf16": RLTConfig("s140m_bf16", 768, 12, 64, 12, 3072, 128, 12, 1.0, 256, 1024,
                            "bf16", 0.02),
    # Reference depth: d=2048, 16 heads x 128, 48 blocks, FFN 8192, W=256, G=1, B=32, T=4096.
    "depth48_bf16": RLTConfig("depth48_bf16", 2048, 16, 128, 48, 8192, 256, 1, 1.0, 32, 4096,
                              "bf16", 0.01),
    # Long-context ablation pair at 140M scale, G=1, B=16, T=8192, alpha=1 and exactly 0.
    "long_a1_bf16": RLTConfig("long_a1_bf16", 768, 12, 64, 12, 3072, 128, 1, 1.0, 16, 8192,
                              "bf16", 0.02),
    "long_a0_bf16": RLTConfig("long_a0_bf16", 768, 12, 64, 12, 3072, 128, 1, 0.0, 16, 8192,
                              "bf16", 0.02),
}

# Per-layer matrices in the order their stream ids are assigned. Shapes are [in, out]
# (row vector times matrix), except that every name maps to one [L, in, out] array.
MATRIX_NAMES = ("wq", "wk", "wv", "wo", "wcq", "wco", "w1", "w3", "w2")

_ID_S_STAR, _ID_W_GATE, _ID_B_GATE, _ID_GAMMA = 0, 1, 2, 3
_ID_LAYER0 = 16
_ID_GROUP0 = 1 << 20
_ID_E0 = 1 << 24
_HEAD_NAMES = ("embed", "enc_gamma", "enc_gamma_out", "out_gamma", "w_out")
_ID_HEAD0 = 1 << 28
_ID_TOKENS0 = 1 << 29
_ID_UNIFORM0 = 1 << 30


def tensor_id(name: str, index: int = 0) -> int:
    """Stream id of a tensor. ``index`` is the layer, group or sequence number."""
    if name == "s_star":
        return _ID_S_STAR
    if name == "w_gate":
        return _ID_W_GATE
    if name == "b_gate":
        return _ID_B_GATE
    if name == "gamma":
        return _ID_GAMMA
    if name in MATRIX_NAMES:
        return _ID_LAYER0 + 16 * index + MATRIX_NAMES.index(name)
    if name == "wmk":
        return _ID_GROUP0 + 2 * index
    if name == "wmv":
        return _ID_GROUP0 + 2 * index + 1
    if name == "e":
        return _ID_E0 + index
    if name in _HEAD_NAMES:
        return _ID_HEAD0 + _HEAD_NAMES.index(name)
    if name == "tokens":
        return _ID_TOKENS0 + index
    if name == "u":
        return _ID_UNIFORM0 + index
    raise KeyError(name)


def _normal(seed: int, tid: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return x


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); result is float32.

    Storage-format conversion only (finite inputs): keeps the top 16 bits of the float32
    pattern after adding half an ulp of bf16 with the round-half-even correction.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_params(cfg: RLTConfig, seed: int = 0, random_gains: bool = False,
                random_gate_bias: bool = False) -> dict[str, np.ndarray]:
    """All decoder parameters as float32 arrays (bf16-representable for bf16 configs).

    Keys and shapes (math convention ``y = x @ W``):
      s_star [d]            learned start state, N(0, 1), never rounded (the state is fp32)
      w_gate [2d, d]        gate over the concatenation [e_t ; alpha * s_{t-1}]
      b_gate [d]            gate bias, zero unless ``random_gate_bias``
      gamma  [L, 3, d]      RMSNorm gains before self-attention, cross-attention and FFN;
                            ones unless ``random_gains`` (then 1 + 0.1 N(0, 1))
      wq wk wv wo wcq wco   [L, d, d]
      w1 w3 [L, d, F], w2 [L, F, d]
      wmk wmv [G, d, d]     memory key/value projections of the encoder outputs
    Matrices are N(0, sigma).
    """
    d, L, F, G = cfg.d, cfg.n_layers, cfg.ffn, cfg.n_groups
    jobs = {"s_star": (tensor_id("s_star"), (d,), 1.0),
            "w_gate": (tensor_id("w_gate"), (2 * d, d), cfg.sigma)}
    for l in range(L):
        for name in MATRIX_NAMES:
            shape = (d, F) if name in ("w1", "w3") else (F, d) if name == "w2" else (d, d)
            jobs[(name, l)] = (tensor_id(name, l), shape, cfg.sigma)
    for g in range(G):
        jobs[("wmk", g)] = (tensor_id("wmk", g), (d, d), cfg.sigma)
        jobs[("wmv", g)] = (tensor_id("wmv", g), (d, d), cfg.sigma)
    rounding = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)

    def run(item):
        key, (tid, shape, std) = item
        x = _normal(seed, tid, shape, std)
        return key, (x if key == "s_star" else rounding(x))

    with ThreadPoolExecutor(_workers()) as ex:
        out = dict(ex.map(run, jobs.items()))
    p = {"s_star": out.pop("s_star"), "w_gate": out.pop("w_gate")}
    p["b_gate"] = (_normal(seed, tensor_id("b_gate"), (d,), 0.5) if random_gate_bias
                   else np.zeros(d, np.float32))
    p["gamma"] = ((1.0 + _normal(seed, tensor_id("gamma"), (L, 3, d), 0.1)).astype(np.float32)
                  if random_gains else np.ones((L, 3, d), np.float32))
    for name in MATRIX_NAMES:
        p[name] = np.stack([out.pop((name, l)) for l in range(L)])
    p["wmk"] = np.stack([out.pop(("wmk", g)) for g in range(G)])
    p["wmv"] = np.stack([out.pop(("wmv", g)) for g in range(G)])
    return p


def make_encoder_outputs(cfg: RLTConfig, seqs, seq_len: int | None = None,
                         seed: int = 0) -> np.ndarray:
    """Encoder outputs e [len(seqs), T, d] ~ N(0, 1) for the listed sequence numbers.

    Sequence b always gets the same values whatever else is requested, so a subset of the
    batch can be regenerated alone. bf16 configs round to bf16.
    """
    T = cfg.seq_len if seq_len is None else int(seq_len)
    seqs = list(seqs)
    out = np.empty((len(seqs), T, cfg.d), np.float32)

    def run(i):
        x = _normal(seed, tensor_id("e", seqs[i]), (T, cfg.d), 1.0)
        out[i] = round_bf16(x) if cfg.dtype == "bf16" else x

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, range(len(seqs))))
    return out


def make_head_params(cfg: RLTConfig, vocab: int = VOCAB, seed: int = 0,
                     random_gains: bool = False) -> dict[str, np.ndarray]:
    """Parameters of the encoder and the readout around the decoder (float32 arrays,
    bf16-representable matrices for bf16 configs). The encoder's attention and FFN matrices
    are the decoder's (make_params), so only these are new:
      embed [V, d]             token embedding, N(0, 1)
      enc_gamma [L, 2, d]      encoder RMSNorm gains before attention and FFN
      enc_gamma_out [d]        gain of the norm that gives e_t
      out_gamma [d]            gain of the readout's norm of s_t
      w_out [d, V]             readout matrix, N(0, sigma)
    Gains are ones unless ``random_gains`` (then 1 + 0.1 N(0, 1))."""
    d, L = cfg.d, cfg.n_layers
    rounding = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)

    def gains(name, shape):
        if not random_gains:
            return np.ones(shape, np.float32)
        return (1.0 + _normal(seed, tensor_id(name), shape, 0.1)).astype(np.float32)

    return {"embed": rounding(_normal(seed, tensor_id("embed"), (vocab, d), 1.0)),
            "enc_gamma": gains("enc_gamma", (L, 2, d)),
            "enc_gamma_out": gains("enc_gamma_out", (d,)),
            "out_gamma": gains("out_gamma", (d,)),
            "w_out": rounding(_normal(seed, tensor_id("w_out"), (d, vocab), cfg.sigma))}


def make_tokens(seqs, seq_len: int, vocab: int = VOCAB, seed: int = 0) -> np.ndarray:
    """Token ids [len(seqs), seq_len] (int32), uniform over the vocabulary, one stream per
    sequence number."""
    out = np.empty((len(list(seqs)), seq_len), np.int32)
    for i, b in enumerate(seqs):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id(
            "tokens", b)])))
        out[i] = rng.integers(0, vocab, seq_len, dtype=np.int32)
    return out


def make_uniforms(n: int, step: int = 0, seed: int = 0) -> np.ndarray:
    """n uniform draws in [0, 1) (float32) for the sampler's step `step`."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id(
        "u", step)])))
    return rng.random(n, dtype=np.float32)
