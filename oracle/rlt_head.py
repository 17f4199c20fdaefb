"""CPU oracle of the encoder that feeds the decoder and of the readout/sampler that follows it.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module: only the tests, the package's smoke check and the benchmark's CPU-baseline leg use
it. It shares no code with the HIP path.

What is computed, and where it is described:

* "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section "Architecture:
  encoder memory meets recurrent decoder": a causal encoder processes the tokens in parallel
  under a causal mask and produces the representations e_t that the memory is projected from
  and that the gated merge reads; the next-token distribution is read from s_t. In the
  reference tied configuration the encoder has as many layers as the decoder, and compatible
  attention and FFN weights are shared between them.
* The same page, section "Three design principles and their caveats" (model-RL co-design): the
  sampler records every action's behaviour log-probability under the distribution it actually
  sampled from, temperature and truncation included.

The pages give no formulas for either part. The readings taken here (each with its reason in
the repository's design notes):
  embedding  x_0 = E[token] (a [V, d] table), no positional encoding (as in the decoder)
  encoder    block l = pre-RMSNorm causal self-attention over positions 1..t, then pre-RMSNorm
             SiLU-gated FFN, both residual, with the decoder block l's matrices
             (W_q, W_k, W_v, W_o, W_1, W_3, W_2) and the encoder's own gains; e_t = RMSNorm of
             the last block's output with a final gain
  readout    logits_t = RMSNorm(s_t; gamma_out) W_out, W_out [d, V]
  sampler    q = softmax(logits / temperature). Order the tokens by descending q, ties by
             ascending token id. Top-k keeps the first k of that order (k = 0 or k >= V: all).
             Top-p keeps the shortest prefix of that order, among the top-k tokens, whose mass
             reaches p times the top-k mass (p >= 1: all of them). pi = q on the kept set,
             renormalised. The action is the first kept token, in ascending token id, at which
             the running sum of pi exceeds u (u uniform in [0, 1), given as input); if rounding
             leaves every running sum <= u, the last kept token. Temperature 0 is greedy: the
             first maximal logit, with probability 1. Recorded: the action, its behaviour
             log-probability log pi(action), and the model's own log-probability
             log softmax(logits)(action) at temperature 1 without truncation.

All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from .rlt_oracle import prepare_params, rms_norm, silu

__all__ = ["embed", "causal_self_attention", "encode", "readout_logits", "log_softmax",
           "kept_tokens", "sample", "sample_rows"]


def embed(head: dict, tokens: np.ndarray) -> np.ndarray:
    """x_0 [B, n, d] = rows of the embedding table E [V, d] at the token ids [B, n]."""
    return np.asarray(head["embed"], np.float64)[np.asarray(tokens)]


def causal_self_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          n_heads: int) -> np.ndarray:
    """Multi-head attention of every position over positions 1..t of the same sequence.

    q, k, v [B, n, d]; per head (contiguous hd = d / n_heads features) the query at position
    t weighs keys 1..t by softmax(q . k / sqrt(hd)) (max subtracted) and sums the values.
    """
    B, n, d = q.shape
    hd = d // n_heads
    out = np.empty((B, n, d))
    for t in range(n):
        for h in range(n_heads):
            sl = slice(h * hd, (h + 1) * hd)
            sc = np.einsum("bk,bjk->bj", q[:, t, sl], k[:, :t + 1, sl]) / np.sqrt(hd)
            sc = sc - sc.max(axis=-1, keepdims=True)
            w = np.exp(sc)
            w = w / w.sum(axis=-1, keepdims=True)
            out[:, t, sl] = np.einsum("bj,bjk->bk", w, v[:, :t + 1, sl])
    return out


def encode(params: dict, head: dict, cfg, tokens: np.ndarray) -> np.ndarray:
    """Encoder outputs e [B, n, d] of the token ids [B, n] (token-parallel, causal).

    Block l runs x += Attn(RMSNorm(x; g_l0)) W_o[l] over positions 1..t, then
    x += (SiLU(f W_1[l]) * (f W_3[l])) W_2[l] with f = RMSNorm(x; g_l1), reusing the decoder
    block l's matrices; e = RMSNorm(x; g_out) after the last block.
    """
    p = prepare_params(params)
    hd_ = prepare_params(head)
    x = embed(hd_, tokens)
    for l in range(cfg.n_layers):
        g = hd_["enc_gamma"][l]
        a = rms_norm(x, g[0], cfg.eps)
        q, k, v = a @ p["wq"][l], a @ p["wk"][l], a @ p["wv"][l]
        x = x + causal_self_attention(q, k, v, cfg.n_heads) @ p["wo"][l]
        f = rms_norm(x, g[1], cfg.eps)
        x = x + (silu(f @ p["w1"][l]) * (f @ p["w3"][l])) @ p["w2"][l]
    return rms_norm(x, hd_["enc_gamma_out"], cfg.eps)


def readout_logits(head: dict, cfg, s: np.ndarray) -> np.ndarray:
    """Next-token logits [B, V] read from the decoder outputs s [B, d]."""
    h = prepare_params(head)
    return rms_norm(np.asarray(s, np.float64), h["out_gamma"], cfg.eps) @ h["w_out"]


def log_softmax(z: np.ndarray) -> np.ndarray:
    """log softmax over the last axis, max subtracted."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True))


def _descending_order(q: np.ndarray) -> np.ndarray:
    # descending probability, ties by ascending token id (a stable sort of -q keeps id order)
    return np.argsort(-q, kind="stable")


def kept_tokens(logits: np.ndarray, temperature: float, top_k: int, top_p: float):
    """(kept mask [V], q [V]) of one row: q = softmax(logits / temperature) and the tokens
    that survive top-k then top-p truncation (temperature > 0)."""
    z = np.asarray(logits, np.float64) / temperature
    q = np.exp(z - z.max())
    q = q / q.sum()
    V = q.shape[0]
    order = _descending_order(q)
    k = V if top_k <= 0 or top_k >= V else int(top_k)
    top = order[:k]
    keep = np.zeros(V, bool)
    if top_p >= 1.0:
        keep[top] = True
        return keep, q
    target = top_p * q[top].sum()
    run = 0.0
    for i in top:
        keep[i] = True
        run += q[i]
        if run >= target:
            break
    return keep, q


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float):
    """One row: (action, behaviour log-probability, model log-probability, kept mask)."""
    logits = np.asarray(logits, np.float64)
    model_lp = log_softmax(logits)
    if temperature == 0.0:
        a = int(np.argmax(logits))  # first maximal entry
        keep = np.zeros(logits.shape[0], bool)
        keep[a] = True
        return a, 0.0, float(model_lp[a]), keep
    keep, q = kept_tokens(logits, temperature, top_k, top_p)
    mass = q[keep].sum()
    idx = np.flatnonzero(keep)  # ascending token id
    pi = q[idx] / mass
    run = 0.0
    a = int(idx[-1])
    for i, x in zip(idx, pi):
        run += x
        if run > u:
            a = int(i)
            break
    return a, float(np.log(q[a] / mass)), float(model_lp[a]), keep


def sample_rows(logits: np.ndarray, temperature: float, top_k: int, top_p: float,
                u: np.ndarray):
    """sample() for every row of logits [B, V] with its own u[b]: arrays of actions,
    behaviour log-probabilities, model log-probabilities and kept masks."""
    out = [sample(logits[b], temperature, top_k, top_p, float(u[b]))
           for b in range(logits.shape[0])]
    return (np.array([o[0] for o in out], np.int64), np.array([o[1] for o in out]),
            np.array([o[2] for o in out]), np.stack([o[3] for o in out]))
