"""CPU oracle of the Recurrent Looped Transformer decoder transition H_{t-1} -> H_t.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module: only the tests, the package's smoke check and the benchmark's CPU-baseline leg use
it. It shares no code with the HIP path; the only thing both sides share is the seeded
input generator in ``synth``.

What is computed, and where it is described (page titles as given in the source text):

* "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section "Architecture:
  encoder memory meets recurrent decoder": the encoder outputs e_t are projected into a
  key-value memory M_{<=t}, shared by all decoder layers (G = 1) or layer-specific
  (G = L_D). The decoder state is H_t = (s_t, C_t^D): the final decoder output vector and
  the retained sliding-window keys/values of every decoder layer. Per token, a gated merge
  combines e_t with s_{t-1}; then every decoder block runs causal sliding-window
  self-attention over decoder activations, cross-attention to the encoder memory and an
  FFN. The window W counts the current token, so at most W - 1 past entries per layer are
  kept. A learned start state s* and an empty cache initialise the system once, before the
  first token, with no reset later.
* "Recurrent Looped Transformer (RLT): prompts in parallel, depth in sequence", section
  "What is this technology": the memory is prefix-restricted; the decoder passes its final
  hidden state and layer-wise SWA cache between tokens.
* The flowtivity page ("recurrent-looped-transformer-debunked"), section "What is the
  Recurrent Looped Transformer?" (the gated merge takes the current token's encoder
  representation and the previous token's final decoder output), and its section "What
  did the independent evaluation find?" with the promtvault story ("16 per-token
  recurrence, no quality gain") on the feedback scale whose zero setting removes the
  recurrent path.

The pages give no formulas. Where they leave a step open this module takes the plainest
reading (listed with its reasons in the design notes of the repository):
  gate      g = sigmoid([e_t ; alpha s_{t-1}] W_g + b_g),  h = g * e_t + (1 - g) * alpha s_{t-1}
  blocks    pre-RMSNorm residual sublayers in the order SWA -> cross-attention -> FFN
  RMSNorm   gamma * x / sqrt(mean(x^2) + eps)
  FFN       (SiLU(f W_1) * (f W_3)) W_2
  attention multi-head, H * hd = d, no biases, no positional encoding, softmax scale
            1 / sqrt(hd); cross-attention at token t (1-based) sees memory entries 1..t
  s_t       the residual stream after the last block (no final norm)
  memory    K_j = e_j W_mK^(g), V_j = e_j W_mV^(g)

All arithmetic is float64 unless ``dtype`` says otherwise. Arrays carry a leading batch
axis of independent sequences; every sequence is computed as if alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rms_norm", "sigmoid", "silu", "attend", "gate_merge", "memory_projection",
    "OracleState", "init_state", "decoder_step", "run_sequence", "export_caches",
    "prepare_params",
]


# --- elementary functions ------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times a per-feature gain."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-x))."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    return x * sigmoid(x)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, n_heads: int) -> np.ndarray:
    """Multi-head softmax attention of one query per sequence over ``n`` key/value rows.

    q [B, d]; keys, values [B, n, d]; the d features are split into ``n_heads`` contiguous
    heads of d / n_heads. Per head: weights softmax_j(q . k_j / sqrt(hd)) (max subtracted),
    output sum_j weight_j v_j. Heads are concatenated back to [B, d].
    """
    B, n, d = keys.shape
    hd = d // n_heads
    qh = q.reshape(B, n_heads, hd)
    kh = keys.reshape(B, n, n_heads, hd)
    vh = values.reshape(B, n, n_heads, hd)
    scores = np.einsum("bhk,bnhk->bhn", qh, kh) / np.sqrt(hd)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    out = np.einsum("bhn,bnhk->bhk", w, vh)
    return out.reshape(B, d)


# --- the method -----------------------------------------------------------------------------

def prepare_params(params: dict, dtype=np.float64) -> dict:
    """Copy of the parameter dict with every array cast to ``dtype``."""
    return {k: np.asarray(v, dtype=dtype) for k, v in params.items()}


def gate_merge(p: dict, alpha: float, e_t: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
    """Gated merge of the encoder output e_t with the feedback-scaled previous output.

    u = alpha * s_{t-1};  g = sigmoid([e_t ; u] W_g + b_g);  h = g * e_t + (1 - g) * u.
    With alpha = 0 the previous output has no influence at all.
    """
    u = alpha * s_prev
    g = sigmoid(np.concatenate([e_t, u], axis=-1) @ p["w_gate"] + p["b_gate"])
    return g * e_t + (1.0 - g) * u


def memory_projection(p: dict, e: np.ndarray):
    """Token-parallel projection of encoder outputs into memory keys and values.

    e [B, T, d] -> (Km, Vm), each [G, B, T, d]: Km[g] = e W_mK^(g), Vm[g] = e W_mV^(g).
    """
    km = np.stack([e @ p["wmk"][g] for g in range(p["wmk"].shape[0])])
    vm = np.stack([e @ p["wmv"][g] for g in range(p["wmv"].shape[0])])
    return km, vm


@dataclass
class OracleState:
    """Decoder state H_t = (s_t, C_t^D) of a batch of sequences.

    ``cache_k[l]`` / ``cache_v[l]`` list the retained self-attention keys/values of layer l,
    oldest first, each entry [B, d]; never more than W - 1 of them. ``t`` counts processed
    tokens (0 before the first one).
    """
    s: np.ndarray
    cache_k: list = field(default_factory=list)
    cache_v: list = field(default_factory=list)
    t: int = 0


def init_state(p: dict, cfg, batch: int) -> OracleState:
    """s_0 = s* for every sequence, empty caches, t = 0."""
    s = np.broadcast_to(p["s_star"], (batch, cfg.d)).copy()
    return OracleState(s=s, cache_k=[[] for _ in range(cfg.n_layers)],
                       cache_v=[[] for _ in range(cfg.n_layers)], t=0)


def decoder_step(p: dict, cfg, state: OracleState, km: np.ndarray, vm: np.ndarray,
                 e_t: np.ndarray) -> np.ndarray:
    """One recurrent transition for every sequence; mutates ``state`` and returns s_t [B, d].

    ``km``/``vm`` [G, B, >=t, d] hold the memory of tokens 1..t (1-based t = state.t + 1).
    """
    t = state.t + 1
    H = cfg.n_heads
    h = gate_merge(p, cfg.alpha, e_t, state.s)
    for l in range(cfg.n_layers):
        gam = p["gamma"][l]
        # causal sliding-window self-attention: window = retained W-1 entries + current
        a = rms_norm(h, gam[0], cfg.eps)
        q, k, v = a @ p["wq"][l], a @ p["wk"][l], a @ p["wv"][l]
        keys = np.stack(state.cache_k[l] + [k], axis=1)
        vals = np.stack(state.cache_v[l] + [v], axis=1)
        h = h + attend(q, keys, vals, H) @ p["wo"][l]
        # cross-attention to the prefix-restricted memory M_{<=t} of this layer's group
        c = rms_norm(h, gam[1], cfg.eps)
        g = 0 if cfg.n_groups == 1 else l
        h = h + attend(c @ p["wcq"][l], km[g][:, :t], vm[g][:, :t], H) @ p["wco"][l]
        # SiLU-gated feed-forward
        f = rms_norm(h, gam[2], cfg.eps)
        h = h + (silu(f @ p["w1"][l]) * (f @ p["w3"][l])) @ p["w2"][l]
        # retain this token's key/value; keep at most W-1 past entries
        state.cache_k[l].append(k)
        state.cache_v[l].append(v)
        while len(state.cache_k[l]) > cfg.window - 1:
            state.cache_k[l].pop(0)
            state.cache_v[l].pop(0)
    state.s = h
    state.t = t
    return h


def run_sequence(params: dict, cfg, e: np.ndarray, state: OracleState | None = None,
                 dtype=np.float64, memory=None):
    """Run the recurrence over encoder outputs e [B, n, d].

    Starts from ``state`` (default: a fresh s*/empty-cache state) at position state.t, so
    ``e`` holds the tokens state.t+1 .. state.t+n. ``memory`` may pass precomputed (Km, Vm)
    covering at least state.t + n tokens; otherwise it is projected from ``e`` (which then
    must start at token 1). Returns (s_traj [B, n, d], state).
    """
    p = params if params["w_gate"].dtype == dtype else prepare_params(params, dtype)
    e = np.asarray(e, dtype=dtype)
    B, n, _ = e.shape
    if state is None:
        state = init_state(p, cfg, B)
    if memory is None:
        if state.t != 0:
            raise ValueError("memory must be given when continuing from t > 0")
        memory = memory_projection(p, e)
    km, vm = memory
    traj = np.empty((B, n, cfg.d), dtype=dtype)
    for i in range(n):
        traj[:, i] = decoder_step(p, cfg, state, km, vm, e[:, i])
    return traj, state


def export_caches(cfg, state: OracleState):
    """Retained caches in canonical order: (K, V) [L, B, W-1, d], oldest first, zero padded,
    and the number of valid entries min(t, W-1)."""
    L, B, d, keep = cfg.n_layers, state.s.shape[0], cfg.d, max(cfg.window - 1, 0)
    K = np.zeros((L, B, keep, d), state.s.dtype)
    V = np.zeros((L, B, keep, d), state.s.dtype)
    n_valid = min(state.t, keep)
    for l in range(L):
        for i in range(n_valid):
            K[l, :, i] = state.cache_k[l][i]
            V[l, :, i] = state.cache_v[l][i]
    return K, V, n_valid
