"""CPU oracle of the reverse-traversal backward pass (backpropagation through time) of the
Recurrent Looped Transformer decoder.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module: only the tests use it. It shares no code with the HIP path.

What is computed and where it is described:

* "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section "Training and
  serving implications": pretraining backpropagates through the whole sequence; the
  derivative of one state with respect to the previous one has terms that run through the
  decoder's self-attention keys and values, not only through s_t, so a correct backward pass
  carries gradients along both paths.
* "16 per-token recurrence, no quality gain" (promtvault), the section on the training bill:
  the decoder is trained with a backward pass that walks the tokens in reverse.

The forward map is the one in ``rlt_oracle`` (the same readings of the pages). For upstream
gradients G[b, t] = dLoss/ds_t the loss is taken as Loss = sum_{b,t} G[b, t] . s_t(b), so the
gradients returned here are the vector-Jacobian product of the whole sequence map with G.
Every rule below is the chain rule applied to one forward operation, written out:

  linear      y = x W              dx = dy W^T,  dW += x^T dy
  RMSNorm     y = gain * x * r,    r = (mean(x^2) + eps)^(-1/2)
              dx = gain * dy * r - x * r^3 * sum(gain * dy * x) / d,  dgain += dy * x * r
  softmax attention, one head:  p = softmax(q . k_j / sqrt(hd)),  o = sum_j p_j v_j
              dv_j = p_j do,  dp_j = do . v_j,  dz_j = p_j (dp_j - sum_i p_i dp_i)
              dq = sum_j dz_j k_j / sqrt(hd),  dk_j = dz_j q / sqrt(hd)
  SiLU gate   m = silu(u1) * u3:   du1 = dm * u3 * sigma(u1) (1 + u1 (1 - sigma(u1))),
              du3 = dm * silu(u1)
  gated merge h = g e + (1 - g) u,  u = alpha s_{t-1},  g = sigma([e ; u] W_g + b_g)
              dg = dh (e - u),  dz = dg g (1 - g),  [de_gate ; du_gate] = dz W_g^T
              de += dh g + de_gate,  du = dh (1 - g) + du_gate,  ds_{t-1} += alpha du

Walking the tokens from last to first, the gradient of a self-attention key/value of token j
collects the contributions of every later token whose window holds it before token j itself is
reached, so when the walk arrives at token j that gradient is complete and flows back into
the projections of token j. Memory keys/values collect contributions from every token t >= j
and flow back into the memory projection (and so into e_j) at the end.

All arithmetic is float64 unless ``dtype`` says otherwise.
"""
from __future__ import annotations

import numpy as np

from .rlt_oracle import memory_projection, prepare_params, rms_norm, sigmoid, silu

__all__ = ["GRAD_NAMES", "bptt", "sequence_loss"]

# Gradient names: every parameter of the forward map, in the order of its weight struct.
GRAD_NAMES = ("s_star", "w_gate", "b_gate", "gamma", "wq", "wk", "wv", "wo", "wcq", "wco",
              "w1", "w3", "w2", "wmk", "wmv")


def _rms_scale(x, eps):
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rms_norm_backward(x, gain, dy, eps):
    """dx and the per-row contribution to dgain of y = gain * x * r."""
    r = _rms_scale(x, eps)
    d = x.shape[-1]
    inner = np.sum(gain * dy * x, axis=-1, keepdims=True)
    dx = gain * dy * r - x * r ** 3 * inner / d
    return dx, dy * x * r


def _attention_probs(q, keys, n_heads):
    """Per-head softmax weights of one query over n keys: [B, H, n]."""
    B, n, d = keys.shape
    hd = d // n_heads
    qh = q.reshape(B, n_heads, hd)
    kh = keys.reshape(B, n, n_heads, hd)
    z = np.einsum("bhk,bnhk->bhn", qh, kh) / np.sqrt(hd)
    z = z - z.max(axis=-1, keepdims=True)
    w = np.exp(z)
    return w / w.sum(axis=-1, keepdims=True)


def _attention_forward(q, keys, vals, n_heads):
    B, n, d = keys.shape
    p = _attention_probs(q, keys, n_heads)
    o = np.einsum("bhn,bnhk->bhk", p, vals.reshape(B, n, n_heads, d // n_heads))
    return o.reshape(B, d), p


def _attention_backward(q, keys, vals, p, do, n_heads):
    """(dq [B, d], dkeys [B, n, d], dvals [B, n, d]) of o = softmax(q k^T / sqrt(hd)) v."""
    B, n, d = keys.shape
    hd = d // n_heads
    qh = q.reshape(B, n_heads, hd)
    kh = keys.reshape(B, n, n_heads, hd)
    vh = vals.reshape(B, n, n_heads, hd)
    doh = do.reshape(B, n_heads, hd)
    dv = np.einsum("bhn,bhk->bnhk", p, doh)
    dp = np.einsum("bhk,bnhk->bhn", doh, vh)
    dz = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    dq = np.einsum("bhn,bnhk->bhk", dz, kh) / np.sqrt(hd)
    dk = np.einsum("bhn,bhk->bnhk", dz, qh) / np.sqrt(hd)
    return dq.reshape(B, d), dk.reshape(B, n, d), dv.reshape(B, n, d)


def sequence_loss(traj: np.ndarray, G: np.ndarray) -> float:
    """Loss = sum_{b,t} G[b, t] . s_t(b) for a trajectory [B, n, d]."""
    return float(np.sum(np.asarray(traj, np.float64) * np.asarray(G, np.float64)))


def bptt(params: dict, cfg, e: np.ndarray, G: np.ndarray, dtype=np.float64, segment: int = 0,
         detach=()):
    """Forward pass from the start state (s*, empty caches, memory projected from e) over the
    n tokens of e [B, n, d], then the reverse traversal for upstream gradients G [B, n, d].

    Returns (s_traj [B, n, d], grads, de): grads maps every name in GRAD_NAMES to an array of
    that parameter's shape; de [B, n, d] is the gradient with respect to the encoder outputs
    (through the gated merge and through the memory projection).

    Truncation (the training section of the first page asks that every detached tensor be
    named): with segment = k > 0 the tokens form segments [0, k), [k, 2k), ... and at every
    segment start the tensors named in `detach` carry no gradient back into the previous
    segment: "state" = the carried output s (the gated merge's input u), "window" = the
    self-attention keys/values of earlier tokens still inside the window. The memory is never
    detached. Detaching "state" alone leaves the window path open.
    """
    detach = set(detach)
    unknown = detach - {"state", "window"}
    if unknown:
        raise ValueError(f"unknown detached tensors {sorted(unknown)}")
    p = params if params["w_gate"].dtype == dtype else prepare_params(params, dtype)
    e = np.asarray(e, dtype)
    G = np.asarray(G, dtype)
    B, n, d = e.shape
    L, H, W, alpha, eps = cfg.n_layers, cfg.n_heads, cfg.window, cfg.alpha, cfg.eps
    grp = [0 if cfg.n_groups == 1 else l for l in range(L)]
    km, vm = memory_projection(p, e)

    # ---- forward, keeping what the reverse walk needs ---------------------------------------
    s = np.broadcast_to(p["s_star"], (B, d)).copy()
    k_all = [[] for _ in range(L)]  # every token's self-attention key/value, per layer
    v_all = [[] for _ in range(L)]
    tape = []
    traj = np.empty((B, n, d), dtype)
    for t in range(n):  # 0-based token index; the memory prefix is entries 0..t
        u = alpha * s
        xin = np.concatenate([e[:, t], u], axis=-1)
        g = sigmoid(xin @ p["w_gate"] + p["b_gate"])
        h = g * e[:, t] + (1.0 - g) * u
        step = {"s_prev": s, "xin": xin, "g": g, "layers": []}
        for l in range(L):
            gam = p["gamma"][l]
            rec = {"x": h}
            a = rms_norm(h, gam[0], eps)
            q, k, v = a @ p["wq"][l], a @ p["wk"][l], a @ p["wv"][l]
            k_all[l].append(k)
            v_all[l].append(v)
            lo = max(0, t - W + 1)  # window: this token and the W - 1 before it
            keys = np.stack(k_all[l][lo:t + 1], axis=1)
            vals = np.stack(v_all[l][lo:t + 1], axis=1)
            o, pw = _attention_forward(q, keys, vals, H)
            y = h + o @ p["wo"][l]
            c = rms_norm(y, gam[1], eps)
            qc = c @ p["wcq"][l]
            oc, pc = _attention_forward(qc, km[grp[l]][:, :t + 1], vm[grp[l]][:, :t + 1], H)
            z = y + oc @ p["wco"][l]
            f = rms_norm(z, gam[2], eps)
            u1, u3 = f @ p["w1"][l], f @ p["w3"][l]
            m = silu(u1) * u3
            h = z + m @ p["w2"][l]
            rec.update(a=a, q=q, lo=lo, pw=pw, o=o, y=y, c=c, qc=qc, pc=pc, oc=oc, z=z, f=f,
                       u1=u1, u3=u3, m=m)
            step["layers"].append(rec)
        s = h
        traj[:, t] = s
        tape.append(step)

    # ---- reverse traversal ------------------------------------------------------------------
    gr = {name: np.zeros_like(p[name]) for name in GRAD_NAMES}
    de = np.zeros_like(e)
    dkm = np.zeros_like(km)
    dvm = np.zeros_like(vm)
    dk_all = np.zeros((L, B, n, d), dtype)  # gradients of the self-attention keys/values
    dv_all = np.zeros((L, B, n, d), dtype)
    carry = np.zeros((B, d), dtype)  # dLoss/ds_t through token t+1's gated merge
    for t in range(n - 1, -1, -1):
        step = tape[t]
        if segment and "state" in detach and (t + 1) % segment == 0:
            carry = np.zeros_like(carry)  # s_t enters the next segment as a constant
        dh = G[:, t] + carry
        for l in range(L - 1, -1, -1):
            r = step["layers"][l]
            gam = p["gamma"][l]
            # feed-forward sublayer: h = z + (silu(f W1) * (f W3)) W2
            gr["w2"][l] += r["m"].T @ dh
            dm = dh @ p["w2"][l].T
            sg = sigmoid(r["u1"])
            du1 = dm * r["u3"] * sg * (1.0 + r["u1"] * (1.0 - sg))
            du3 = dm * silu(r["u1"])
            gr["w1"][l] += r["f"].T @ du1
            gr["w3"][l] += r["f"].T @ du3
            df = du1 @ p["w1"][l].T + du3 @ p["w3"][l].T
            dz, dgain = _rms_norm_backward(r["z"], gam[2], df, eps)
            gr["gamma"][l, 2] += dgain.sum(axis=0)
            dz = dz + dh
            # cross-attention sublayer: z = y + attend(c Wcq, memory 0..t) Wco
            gr["wco"][l] += r["oc"].T @ dz
            doc = dz @ p["wco"][l].T
            dqc, dkeys, dvals = _attention_backward(
                r["qc"], km[grp[l]][:, :t + 1], vm[grp[l]][:, :t + 1], r["pc"], doc, H)
            dkm[grp[l]][:, :t + 1] += dkeys
            dvm[grp[l]][:, :t + 1] += dvals
            gr["wcq"][l] += r["c"].T @ dqc
            dc = dqc @ p["wcq"][l].T
            dy, dgain = _rms_norm_backward(r["y"], gam[1], dc, eps)
            gr["gamma"][l, 1] += dgain.sum(axis=0)
            dy = dy + dz
            # self-attention sublayer: y = x + attend(a Wq, window keys/values) Wo
            gr["wo"][l] += r["o"].T @ dy
            do = dy @ p["wo"][l].T
            lo = r["lo"]
            keys = np.stack(k_all[l][lo:t + 1], axis=1)
            vals = np.stack(v_all[l][lo:t + 1], axis=1)
            dq, dkeys, dvals = _attention_backward(r["q"], keys, vals, r["pw"], do, H)
            if segment and "window" in detach:
                # keys/values of tokens before this token's segment enter it as constants
                first = (t // segment) * segment
                dkeys[:, :max(0, first - lo)] = 0.0
                dvals[:, :max(0, first - lo)] = 0.0
            dk_all[l][:, lo:t + 1] += dkeys
            dv_all[l][:, lo:t + 1] += dvals
            # every later token that saw this token's key/value has been walked: complete
            dk, dv = dk_all[l][:, t], dv_all[l][:, t]
            gr["wq"][l] += r["a"].T @ dq
            gr["wk"][l] += r["a"].T @ dk
            gr["wv"][l] += r["a"].T @ dv
            da = dq @ p["wq"][l].T + dk @ p["wk"][l].T + dv @ p["wv"][l].T
            dx, dgain = _rms_norm_backward(r["x"], gam[0], da, eps)
            gr["gamma"][l, 0] += dgain.sum(axis=0)
            dh = dx + dy
        # gated merge
        g, xin, u = step["g"], step["xin"], alpha * step["s_prev"]
        dzg = dh * (e[:, t] - u) * g * (1.0 - g)
        gr["w_gate"] += xin.T @ dzg
        gr["b_gate"] += dzg.sum(axis=0)
        dxin = dzg @ p["w_gate"].T
        de[:, t] += dh * g + dxin[:, :d]
        carry = alpha * (dh * (1.0 - g) + dxin[:, d:])
    gr["s_star"] = carry.sum(axis=0)  # s_0 = s* for every sequence
    # memory projection: Km[g] = e WmK[g], Vm[g] = e WmV[g]
    for gi in range(km.shape[0]):
        gr["wmk"][gi] = np.einsum("btd,btk->dk", e, dkm[gi])
        gr["wmv"][gi] = np.einsum("btd,btk->dk", e, dvm[gi])
        de += dkm[gi] @ p["wmk"][gi].T + dvm[gi] @ p["wmv"][gi].T
    return traj, gr, de
